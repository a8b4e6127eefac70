"""Build libpagedkv.so (HIP kernels + C ABI) in-tree for gfx950.

    python -m paged_kv_cache_181_amd.build

Every HIP source is compiled with hipcc for gfx950 only.  Packed-FP32 VALU
instructions are disabled (``-packed-fp32-ops``); divisions stay correctly
rounded (no fast-math), which the bit-exact K8/V4 quantizer relies on.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpagedkv.so")
SOURCES = ["api.hip", "write_kernels.hip", "attn_kernels.hip", "gather_kernels.hip"]
# read-only measurement probes (pagedkv_probe.h), a library of their own
PROBE_LIB = os.path.join(PKG, "libpagedkv_probe.so")
PROBE_SOURCES = ["probe_kernels.hip"]
# measurement variant: the 16-bit partition kernel's scores on vector dot
# products instead of MFMA (same ABI; loaded with PKV_LIBRARY for an A/B)
QKVALU_LIB = os.path.join(PKG, "libpagedkv_qkvalu.so")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source (always, even if the libraries exist) and link the
    decode library and the probe library."""
    _build_lib(SOURCES, LIB, verbose, jobs)
    _build_lib(PROBE_SOURCES, PROBE_LIB, verbose, jobs)
    _build_lib(SOURCES, QKVALU_LIB, verbose, jobs, defines={"attn_kernels.hip": ["-DPKV_QK_VALU=1"]},
               tag="qkvalu")
    return LIB


def _build_lib(sources, lib, verbose, jobs, defines=None, tag=""):
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in sources:
        extra = (defines or {}).get(src, [])
        stem = src.replace(".hip", "") + ("_" + tag if extra else "")
        obj = os.path.join(objdir, stem + ".o")
        objs.append(obj)
        cmd = [cc, *flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    while procs:
        _wait(procs.pop(0))
    tmp = lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if out.returncode != 0:
        raise RuntimeError("link failed:\n" + out.stdout)
    os.replace(tmp, lib)


def _wait(item):
    src, proc = item
    text, _ = proc.communicate()
    text = text.decode(errors="replace")
    # the host pass does not know the packed-fp32 feature; that note is expected
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    rest = "\n".join(l for l in text.splitlines() if noise not in l).strip()
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{rest}")
    if rest:
        print(f"[{src}]\n{rest}", file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
