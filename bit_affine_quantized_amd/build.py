"""Build the HIP library ``libqgemv.so`` for gfx950, in-tree.

The kernels are instantiated per code width in csrc/qgemv_b<bits>.hip and
compiled in parallel with the host code (csrc/qgemv.hip), then linked.
Flags: -ffp-contract=off (every fused operation in the kernels is an explicit
builtin, so no instantiation contracts differently from another), the
packed-fp32 feature switched off for device code, and MFMA results kept in
ordinary VGPRs (the epilogue reads them with plain VALU operands).
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = (["qgemv.hip"] + [f"qgemv_b{b}.hip" for b in (2, 3, 4, 5, 6, 8)]
           + [f"qgemv_wide_b{b}.hip" for b in (2, 3, 4, 5, 6, 8)]
           + [f"qgemv_stack_m{m}.hip" for m in (1, 2, 4, 8, 16)])
LIB = os.path.join(HERE, "libqgemv.so")
BUILD_DIR = os.path.join(HERE, "_build")
# per-kernel registers, scratch, LDS and occupancy, from the compiler's
# resource remarks of the last build
RESOURCES = os.path.join(BUILD_DIR, "kernel_resources.txt")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Rpass-analysis=kernel-resource-usage",
]
_FIELDS = (("VGPRs", "vgprs"), ("AGPRs", "agprs"), ("ScratchSize [bytes/lane]", "scratch"),
           ("Occupancy [waves/SIMD]", "occupancy"), ("VGPRs Spill", "vgpr_spill"),
           ("LDS Size [bytes/block]", "static_lds"))


def _resources(text: str) -> dict:
    """Kernel name -> resource fields, from -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        if cur is None:
            continue
        for label, key in _FIELDS:
            m = re.search(r"remark:\s+" + re.escape(label) + r": (\d+)", line)
            if m:
                out[cur][key] = int(m.group(1))
    return out


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed: {cmd[-3]}")
    return r


def build(out: str = LIB, extra=(), jobs: int | None = None) -> str:
    """Compile every translation unit and link ``out`` (always recompiles)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or max(1, min(len(SOURCES), os.cpu_count() or 1))
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    res = {}
    for r in results:
        res.update(_resources(r.stderr))
    with open(RESOURCES, "w") as f:
        f.write("# kernel vgprs agprs scratch_bytes_per_lane vgpr_spill static_lds occupancy_waves_per_simd\n")
        for name in sorted(res):
            v = res[name]
            f.write(f"{name} {v.get('vgprs', -1)} {v.get('agprs', -1)} {v.get('scratch', -1)} "
                    f"{v.get('vgpr_spill', -1)} {v.get('static_lds', -1)} {v.get('occupancy', -1)}\n")
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
