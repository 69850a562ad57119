"""Build the HIP library ``libqgemv.so`` for gfx950, in-tree.

Flags: -ffp-contract=off (every fused operation in the kernels is an explicit
builtin, so no instantiation contracts differently from another), and the
packed-fp32 feature switched off for device code.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = os.path.join(HERE, "csrc", "qgemv.hip")
LIB = os.path.join(HERE, "libqgemv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-I", os.path.join(ROOT, "include"),
]


def build(out: str = LIB, extra=()) -> str:
    """Compile csrc/qgemv.hip into ``out`` (always recompiles)."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, SOURCE, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libqgemv.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
