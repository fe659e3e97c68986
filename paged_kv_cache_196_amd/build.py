"""Compile the gfx950 library in-tree: csrc/*.hip -> libpagedattn.so.

Every translation unit (the C ABI, the decode kernels per element type and
engine, the prefill kernels per element type, the cache-write and scan
kernels) is compiled to an object in parallel, then linked.  The host-only
timing driver csrc/bm_contend.cpp (block manager under contention) is then
built with the host compiler against the library.

    python -m paged_kv_cache_196_amd.build
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpagedattn.so")
BM_CONTEND = os.path.join(PKG, "bm_contend")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return path


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the online softmax rescales
    # them every sub-tile, which would otherwise shuttle them out of AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]


def compile_command(src: str, obj: str, extra=()) -> list:
    return [hipcc(), *FLAGS, *extra, "-c", src, "-o", obj]


def link_command(objs, out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    return r.returncode, errs


def build(verbose: bool = False, extra=(), jobs: int | None = None) -> str:
    """Compile every source and link the library; return its path.
    extra: additional hipcc flags for the compile steps (e.g. remarks)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in SOURCES]
    cmds = [compile_command(s, o, extra) for s, o in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = [(c, e) for c, (rc, e) in zip(cmds, results) if rc != 0]
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(
            " ".join(c) + "\n" + "\n".join(e) for c, e in failed))
    if verbose:
        for c, (_, e) in zip(cmds, results):
            if e:
                print("\n".join(e), file=sys.stderr)
    tmp = LIB + f".tmp{os.getpid()}"
    rc, errs = _run(link_command(objs, tmp))
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(errs))
    os.replace(tmp, LIB)
    rc, errs = _run(host_tool_command(os.path.join(CSRC, "bm_contend.cpp"), BM_CONTEND))
    if rc != 0:
        raise RuntimeError("bm_contend build failed:\n" + "\n".join(errs))
    return LIB


def resource_usage(jobs: int | None = None) -> dict:
    """Per-kernel resource use of every translation unit, read from the
    compiler's resource-usage remarks (device code only; the objects go to
    a temporary directory).  Returns {kernel symbol: {"VGPRs": n,
    "ScratchSize": bytes per lane, "Occupancy": waves per SIMD, ...}}."""
    import re
    import tempfile

    keys = {"VGPRs": "VGPRs", "AGPRs": "AGPRs", "TotalSGPRs": "SGPRs",
            "ScratchSize [bytes/lane]": "ScratchSize", "Occupancy [waves/SIMD]": "Occupancy",
            "VGPRs Spill": "VGPRSpill", "SGPRs Spill": "SGPRSpill", "LDS Size [bytes/block]": "LDS"}
    with tempfile.TemporaryDirectory() as tmp:
        cmds = [[hipcc(), *FLAGS, "--offload-device-only", "-Rpass-analysis=kernel-resource-usage",
                 "-c", src, "-o", os.path.join(tmp, os.path.basename(src) + ".o")] for src in SOURCES]
        jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds))
    usage = {}
    for cmd, r in zip(cmds, results):
        if r.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + r.stderr[-3000:])
        cur = None
        for line in r.stderr.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = usage.setdefault(m.group(1), {})
                continue
            m = re.search(r"remark: +([A-Za-z][^:]*?): (\d+) \[", line)
            if m and cur is not None and m.group(1) in keys:
                cur[keys[m.group(1)]] = int(m.group(2))
    return usage


def host_tool_command(src: str, out: str) -> list:
    """A host program that calls the library's C entry points (no device
    code of its own), linked to libpagedattn.so beside it."""
    cxx = shutil.which("g++") or shutil.which("c++") or "g++"
    return [cxx, "-O2", "-std=c++17", "-pthread", "-I", INCLUDE, src, "-o", out,
            "-L", PKG, "-lpagedattn", "-Wl,-rpath,$ORIGIN"]


if __name__ == "__main__":
    print(build(verbose=True))
