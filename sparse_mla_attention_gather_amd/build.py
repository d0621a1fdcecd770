"""Build the gfx950 HIP library ``libdsa_mi355x.so`` in-tree with hipcc.

    python -m sparse_mla_attention_gather_amd.build

Every .hip file under ``csrc/`` goes into one shared library exporting the C
ABI of ``include/dsa.h``.  Packed fp32 instructions are disabled for all
device code (``-packed-fp32-ops``); hipcc's host pass warns that it does not
know that feature, which is harmless.

The build fails if any kernel uses scratch memory (spilled vector registers
or stack):
the attention kernel waits for its tile copies by counting outstanding vector
memory operations, which is only right when nothing else (such as a spill)
is in flight.

Each source compiles to its own object (in parallel), so that a file can
carry flags of its own: the attention kernels are built without NaN
semantics (``-fno-honor-nans``), which lets ``fmaxf`` on values read from LDS
or from lane swaps compile to one ``v_max_f32`` instead of two quieting
maxima and one (their inputs are finite scores, -inf for masked entries, or
the finite "no maximum yet" value; pool rows hold finite codes).  The writer
and the query cast keep IEEE NaN handling: they encode NaN inputs.
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
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# flags of single sources (by file name)
FILE_FLAGS = {"attn.hip": ["-fno-honor-nans"]}
# per-kernel resource report (registers, spills, scratch) on stderr
REPORT = ["-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics"]


def scratch_users(report: str):
    """Kernels whose resource report shows scratch memory: a nonzero scratch
    size or spilled vector registers.  (Scalar registers spilled into lanes
    of vector registers, with no scratch, issue no memory operations.)"""
    bad, name = [], None
    for ln in report.splitlines():
        if "Function Name:" in ln:
            name = ln.split("Function Name:")[1].split()[0]
        for key in ("VGPRs Spill:", "ScratchSize [bytes/lane]:"):
            if key in ln and name:
                val = int(ln.split(key)[1].split()[0])
                if val:
                    bad.append((name, key.rstrip(":"), val))
    return bad


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out: str = LIB, defines=(), verbose: bool = False) -> str:
    tmp = out + ".objs"
    os.makedirs(tmp, exist_ok=True)
    jobs = []
    for src in sources():
        base = os.path.basename(src)
        obj = os.path.join(tmp, base + ".o")
        cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(base, []), *REPORT,
               *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((cmd, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.PIPE, text=True)))
    objs, report, failed = [], [], False
    for cmd, obj, proc in jobs:
        _, err = proc.communicate()
        errs = [ln for ln in err.splitlines()
                if "packed-fp32-ops" not in ln and "not a recognized feature" not in ln
                and "kernel-resource-usage" not in ln]
        if proc.returncode != 0:
            sys.stderr.write("\n".join(errs) + "\n")
            failed = True
        elif verbose and errs:
            sys.stderr.write("\n".join(errs) + "\n")
        report.append(err)
        objs.append(obj)
    if failed:
        raise RuntimeError("hipcc failed")
    bad = scratch_users("\n".join(report))
    if bad:
        raise RuntimeError(f"kernels use scratch memory: {bad}")
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise RuntimeError(f"link failed ({res.returncode})")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
