"""Build the HIP library in-tree: ``paged_kv_cache_141_amd/_lib/libpa.so``.

Usage: ``python -m paged_kv_cache_141_amd.build`` (or ``__graft_entry__.build()``).
Always recompiles.  Cross-compiles for gfx950 on a host without a GPU.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libpa.so")
# the same sources with -DPA_DEBUG=1: metadata, block-id and slot checks that
# record the first violation (pa_debug_check) instead of reading out of bounds
DEBUG_LIB = os.path.join(OUT_DIR, "libpa_debug.so")
SOURCES = ["pa_api.hip", "pa_noalloc.hip", "pa_cache_write.hip", "pa_blocks.hip", "pa_metadata.hip", "pa_attention.hip", "pa_decode.hip", "pa_chunk.hip", "pa_step.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: no AGPR<->VGPR copies around the softmax
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # IEEE fp32 division (the fp8 cache write divides by the scale)
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math", "-ffp-contract=fast",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def _scratch_kernels(stderr: str):
    """Kernels whose resource remarks report scratch (spilled registers or a
    stack): (name, bytes per lane)."""
    out, name = [], None
    for line in stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "remark:")
    err = "\n".join(l for l in (r.stderr or "").splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    # No kernel may spill: every kernel is sized to keep its state in
    # registers, and a spilling build of a persistent decode kernel (head dim
    # 256 at half a SIMD's registers) once took the GPU down.
    spilled = _scratch_kernels(r.stderr or "") if RESOURCE_REMARKS in cmd else []
    if spilled:
        raise RuntimeError("kernels use scratch memory (register spills): " +
                           ", ".join(f"{n} ({b} B/lane)" for n, b in spilled))
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile the library to ``out`` (``-D`` ``defines`` override kernel tunables).

    Each source compiles to its own object, in parallel; then one link."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    objdir = out + ".obj"
    os.makedirs(objdir, exist_ok=True)
    common = [hipcc(), *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"),
              "-I", CSRC]
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    jobs = [[*common, RESOURCE_REMARKS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as pool:
        list(pool.map(lambda c: _run(c, verbose), jobs))
    tmp = out + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    shutil.rmtree(objdir, ignore_errors=True)
    return out


# The host validation layer (the C ABI's argument checks, workspace sizing
# and launch arguments) with AddressSanitizer and UndefinedBehaviorSanitizer,
# linked against the stub launchers of tests/host_check instead of the
# kernels: a CPU executable.  The sanitizers instrument host code only.
HOST_CHECK = os.path.join(OUT_DIR, "host_check")
HOST_CHECK_SRC = os.path.join(ROOT, "tests", "host_check", "host_check.cpp")
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_check(verbose: bool = False, out: str = HOST_CHECK) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    objdir = out + ".obj"
    os.makedirs(objdir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f not in ("-O3", "-fPIC")] + ["-O1", "-g"]
    common = [hipcc(), *flags, *SANITIZE, "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = [os.path.join(CSRC, "pa_api.hip"), os.path.join(CSRC, "pa_noalloc.hip"), HOST_CHECK_SRC]
    objs = [os.path.join(objdir, os.path.basename(s).rsplit(".", 1)[0] + ".o") for s in srcs]
    with ThreadPoolExecutor(len(srcs)) as pool:
        list(pool.map(lambda so: _run([*common, "-c", so[0], "-o", so[1]], verbose), zip(srcs, objs)))
    _run([hipcc(), "--offload-arch=gfx950", *SANITIZE, *objs, "-o", out], verbose)
    shutil.rmtree(objdir, ignore_errors=True)
    return out


def build_all(verbose: bool = False):
    """The release library and the debug-checked one, side by side."""
    with ThreadPoolExecutor(2) as pool:
        jobs = [pool.submit(build, verbose, LIB), pool.submit(build, verbose, DEBUG_LIB, ("PA_DEBUG=1",))]
        return [j.result() for j in jobs]


if __name__ == "__main__":
    print(build_all(verbose=True))
