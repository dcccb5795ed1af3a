"""Compile the HIP sources of the TTT inner loop into one in-tree shared library.

    python -m test_long_context_chunk_amd.build

Always recompiles. Needs hipcc (ROCm) but no GPU: gfx950 code is cross-compiled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libttt_mi355x.so"
SOURCES = ["kernels.hip", "gemm_inst.hip", "attention.hip", "ttt_api.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 instructions are kept out of the generated code; the host pass warns
    # that it does not know the feature, which is harmless.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def lib_path() -> str:
    return os.path.join(HERE, LIB_NAME)


def build(verbose: bool = True) -> str:
    out = lib_path()
    objs = []
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    t0 = time.time()
    procs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = False
    for cmd, p in procs:
        text = p.communicate()[0].decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed = True
            sys.stderr.write(" ".join(cmd) + "\n" + text + "\n")
        elif verbose and text.strip():
            sys.stderr.write(text + "\n")
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = out + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} in {time.time() - t0:.1f}s")
    return out


if __name__ == "__main__":
    build()
