"""Build liblrscan.so (HIP, gfx950 only) in-tree.

Every ``csrc/*.hip`` file is compiled by hipcc for gfx950 into an object and
the objects are linked into ``liblrscan.so`` next to this file.  Only the
symbols marked LRSCAN_API in ``include/lrscan.h`` are exported.

``measure/stream_ceiling.hip`` is built the same way into
``libstreamceil.so``: plain streaming kernels with the scan's access
patterns, which only the benchmark loads (the achievable-bandwidth ceiling it
reports beside the scan).

    python -m linear_recurrence_sequence_diag_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblrscan.so")
MEASURE = os.path.join(HERE, "measure")
CEILING_LIB = os.path.join(HERE, "libstreamceil.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed-fp32 instructions in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # arithmetic exactly as written: no implicit multiply-add contraction, so
    # two code paths that spell out the same operations round identically
    "-ffp-contract=off",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *HIP_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link liblrscan.so and libstreamceil.so.
    Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    ceiling_src = os.path.join(MEASURE, "stream_ceiling.hip")
    workers = min(len(srcs) + 1, max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs + [ceiling_src]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], CEILING_LIB)
    if verbose:
        print(f"built {LIB} and {CEILING_LIB}")
    return LIB


if __name__ == "__main__":
    build()
