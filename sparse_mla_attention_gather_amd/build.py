"""Build the gfx950 HIP library ``libdsa_mi355x.so`` in-tree with hipcc.

    python -m sparse_mla_attention_gather_amd.build

Every .hip file under ``csrc/`` goes into one shared library exporting the C
ABI of ``include/dsa.h``.  Packed fp32 instructions are disabled for all
device code (``-packed-fp32-ops``); hipcc's host pass warns that it does not
know that feature, which is harmless.

The build fails if any kernel uses scratch memory (register spills or stack):
the attention kernel waits for its tile copies by counting outstanding vector
memory operations, which is only right when nothing else (such as a spill)
is in flight.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# per-kernel resource report (registers, spills, scratch) on stderr
REPORT = ["-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics"]


def scratch_users(report: str):
    """Kernels whose resource report shows spills or a nonzero scratch size."""
    bad, name = [], None
    for ln in report.splitlines():
        if "Function Name:" in ln:
            name = ln.split("Function Name:")[1].split()[0]
        for key in ("VGPRs Spill:", "SGPRs Spill:", "ScratchSize [bytes/lane]:"):
            if key in ln and name:
                val = int(ln.split(key)[1].split()[0])
                if val:
                    bad.append((name, key.rstrip(":"), val))
    return bad


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out: str = LIB, defines=(), verbose: bool = False) -> str:
    cmd = [HIPCC, *FLAGS, *REPORT, *[f"-D{d}" for d in defines], *sources(),
           "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines()
            if "packed-fp32-ops" not in ln and "not a recognized feature" not in ln
            and "kernel-resource-usage" not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(errs) + "\n")
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    bad = scratch_users(res.stderr)
    if bad:
        os.remove(out + ".tmp")
        raise RuntimeError(f"kernels use scratch memory: {bad}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
