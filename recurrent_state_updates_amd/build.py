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

# (source, object name, extra defines): the kernel instantiation units are
# compiled once per (operator, key width), so that they build in parallel.
# NO_KERNELS: HIP sources that define device data but no kernel, so the
# compiler prints no resource remarks for them.
OPS = {0: "gdn", 1: "kda", 2: "rwkv6"}
KEY_WIDTHS = (32, 64, 128)
SOURCES = [("deltalog.cpp", "deltalog", []), ("slots.hip", "slots", []), ("probe.hip", "probe", []),
           ("static_prep.hip", "static_prep", [])] + [
    (f"kernels_{kind}.hip", f"kernels_{kind}_{OPS[op]}_dk{dk}", [f"-DDLK_OP={op}", f"-DDLK_DK={dk}"])
    for kind in ("step", "chunk") for op in OPS for dk in KEY_WIDTHS]
NO_KERNELS = {"static_prep"}

# Packed fp32 VALU ops are switched off for all device code; the host pass
# prints that it does not know the feature, which is harmless.  Matrix-core
# accumulators are kept in ordinary VGPRs: gfx950 has one register file for
# both kinds, and accumulators in AGPRs would cost a wave of occupancy.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-I", os.path.join(ROOT, "include")]


def _extra_flags():
    """Extra hipcc flags from DELTALOG_HIPCC_FLAGS (space-separated), for
    building variants of the kernels' compile-time knobs (such as
    -DDLK_MIN_WAVES=4) to measure against the default."""
    return os.environ.get("DELTALOG_HIPCC_FLAGS", "").split()


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
    """Raise if a kernel of ``src`` spills VGPRs or uses per-lane scratch.

    Every kernel's remark block must be present and complete: a source that
    yields no block, or a block without both the spill count and the scratch
    size, stops the build too (a toolchain that renamed the fields or stopped
    forwarding the remarks would otherwise pass the guard without checking
    anything).  Returns {kernel: {field: value}} for the blocks found."""
    blocks, fn = {}, None
    for ln in lines:
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            fn = m.group(1)
            blocks.setdefault(fn, {})
            continue
        m = re.search(r"(VGPRs Spill|ScratchSize \[bytes/lane\]|VGPRs|Occupancy \[waves/SIMD\]): (\d+)", ln)
        if m and fn is not None:
            blocks[fn][m.group(1)] = int(m.group(2))
    if not blocks:
        raise RuntimeError(f"{src}: the compiler printed no kernel resource remarks; "
                           "the no-spill guard cannot check this source")
    incomplete = [k for k, f in blocks.items() if "VGPRs Spill" not in f or "ScratchSize [bytes/lane]" not in f]
    if incomplete:
        raise RuntimeError(f"{src}: resource remarks without a spill count or a scratch size for:\n"
                           + "\n".join(incomplete))
    bad = [f"{k}: VGPRs Spill {f['VGPRs Spill']}, ScratchSize {f['ScratchSize [bytes/lane]']}"
           for k, f in blocks.items() if f["VGPRs Spill"] > 0 or f["ScratchSize [bytes/lane]"] > 0]
    if bad:
        raise RuntimeError(f"{src}: kernels that spill to scratch are not built:\n" + "\n".join(bad))
    return blocks


def _default_jobs():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 4
    return max(1, min(16, n))


def build(verbose: bool = False, jobs: int = None) -> str:
    """Compile and link the library; returns its path."""
    hipcc = _hipcc()
    jobs = jobs or _default_jobs()
    os.makedirs(BUILD_DIR, exist_ok=True)
    # a refused or failed build leaves no library behind to be loaded
    tmp = LIB + ".tmp"
    for path in (LIB, tmp):
        if os.path.exists(path):
            os.remove(path)
    objs, cmds = [], []
    for src, name, defines in SOURCES:
        obj = os.path.join(BUILD_DIR, name + ".o")
        objs.append(obj)
        checked = src.endswith(".hip") and name not in NO_KERNELS
        extra = RESOURCE_REMARKS if checked else []
        cmds.append((name, src, [hipcc, *FLAGS, *_extra_flags(), *defines, *extra, "-c", os.path.join(CSRC, src),
                                 "-o", obj]))
    # the longest units first, so that they do not start last
    order = sorted(cmds, key=lambda c: (not c[0].startswith("kernels_chunk"), not c[0].endswith("dk128")))
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        outs = list(ex.map(lambda c: (c[0], c[1], _run(c[2], verbose)), order))
    for name, src, lines in outs:
        if src.endswith(".hip") and name not in NO_KERNELS:
            check_resources(name, lines)
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
