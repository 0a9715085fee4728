"""Build ``libdeltalog.so`` (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: ``python -m recurrent_state_updates_amd.build`` (or via
``__graft_entry__.build()``).  Compiles every translation unit in parallel
into ``_build/`` at the repository root and links the shared library next to
this file.
"""
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdeltalog.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["deltalog.cpp", "kernels_gdn.hip", "kernels_kda.hip", "kernels_rwkv6.hip", "slots.hip",
           "kernels_gdn_chunk.hip", "kernels_kda_chunk.hip", "kernels_rwkv6_chunk.hip"]

# Packed fp32 VALU ops are switched off for all device code; the host pass
# prints that it does not know the feature, which is harmless.  Matrix-core
# accumulators are kept in ordinary VGPRs: gfx950 has one register file for
# both kinds, and accumulators in AGPRs would cost a wave of occupancy.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-I", os.path.join(ROOT, "include")]


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libdeltalog.so")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in res.stdout.splitlines() if "packed-fp32-ops' is not a recognized" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n" + "\n".join(lines))
    remarks = [ln for ln in lines if "remark:" in ln or ln.startswith(" ") or ln.startswith("In file included")]
    others = [ln for ln in lines if ln not in remarks]
    if verbose and others:
        print("\n".join(others), flush=True)
    return lines


# Device code is compiled with the compiler's resource remarks, and a kernel
# that spills registers to scratch memory is refused: several kernels ask for
# an occupancy that the compiler meets only by allocating tightly, and a
# spilling variant is not one that has been run and tested.
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def check_resources(src, lines):
    """Raise if a kernel of ``src`` spills VGPRs or uses per-lane scratch."""
    fn, bad = None, []
    for ln in lines:
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            fn = m.group(1)
            continue
        m = re.search(r"(VGPRs Spill|ScratchSize \[bytes/lane\]): (\d+)", ln)
        if m and int(m.group(2)) > 0:
            bad.append(f"{fn}: {m.group(1)} {m.group(2)}")
    if bad:
        raise RuntimeError(f"{src}: kernels that spill to scratch are not built:\n" + "\n".join(bad))


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile and link the library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        extra = RESOURCE_REMARKS if src.endswith(".hip") else []
        cmds.append((src, [hipcc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        outs = list(ex.map(lambda sc: (sc[0], _run(sc[1], verbose)), cmds))
    for src, lines in outs:
        if src.endswith(".hip"):
            check_resources(src, lines)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
