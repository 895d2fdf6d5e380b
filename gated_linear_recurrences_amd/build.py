"""Build the HIP library ``libglr.so`` in-tree for gfx950.

Every ``csrc/*.hip`` and ``csrc/*.cpp`` file is compiled by hipcc (in parallel)
and linked into ``gated_linear_recurrences_amd/libglr.so``. Run as
``python -m gated_linear_recurrences_amd.build`` or call ``build()``.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libglr.so")
ARCH = "gfx950"


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU ops are kept out of generated code on this target
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in VGPRs: with AGPR accumulators every VALU touch of the carried
        # memory (its bf16 operand, its decay) costs a copy each way
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + _flags() + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in res.stderr.splitlines() if noise not in l).strip()
    return obj, warn


def build(verbose=True):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_compile, srcs))
    for obj, warn in results:
        if warn and verbose:
            print(f"[build] {os.path.basename(obj)}:\n{warn}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] wrote {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
