"""Build the HIP library libgdr.so in-tree for gfx950 with hipcc.

    python -m gated_delta_rule_68_amd.build      # or build() from Python

Every .hip file under csrc/ is compiled to an object (in parallel) and linked
into gated_delta_rule_68_amd/libgdr.so.  Device code is compiled with packed
fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgdr.so")
PROBE_LIB = os.path.join(HERE, "libgdr_probe.so")
ARCH = os.environ.get("GDR_OFFLOAD_ARCH", "gfx950")

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-file additions.  The two-launch KDA chain keeps its state tiles in
# ordinary VGPRs as matrix-core accumulators (gfx950 allows either register
# file): the state is scaled by the decays on the vector ALUs every chunk, and
# in the accumulation registers each of those passes cost two moves per
# element (measured: chain 282-303 us -> 251 us on the prefill layer).
FILE_FLAGS = {
    "kda_prep_chain.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the rate probe: accumulators stay in the VGPRs the products write, so
    # its loop is matrix instructions only
    "mfma_peak.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libgdr.so")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *CXXFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    """Compile every csrc/*.hip and link libgdr.so (and csrc/probe/*.hip into
    libgdr_probe.so, the benchmark's matrix-core rate probe); returns the
    path of libgdr.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probes = sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))
    workers = max(1, min(len(srcs) + len(probes), os.cpu_count() or 1, 8))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs + probes))
    _link(objs[:len(srcs)], LIB)
    if probes:
        _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources for {ARCH}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
