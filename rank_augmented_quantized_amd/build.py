"""Build the HIP library ``libtq.so`` in-tree for gfx950 with hipcc.

Run as ``python -m rank_augmented_quantized_amd.build`` (or call
``build()``); every call recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtq.so")
SOURCES = ["tq_api.hip", "tq_quant.hip", "tq_gemm.hip", "tq_gemm8.hip", "tq_decode.hip", "tq_rht.hip", "tq_qlr.hip", "tq_asym.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or put hipcc on PATH")


def compile_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # floating-point operations exactly as written (fused only where fmaf says so)
        "-ffp-contract=off",
        # no packed fp32 VALU instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE,
    ]


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="tq_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [hipcc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, cmd, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
            if p.returncode != 0:
                failed.append((src, text))
            elif verbose and text.strip():
                print(text)
        if failed:
            msg = "\n".join(f"--- {s} ---\n{t}" for s, t in failed)
            raise RuntimeError(f"hipcc failed:\n{msg}")
        tmp_lib = os.path.join(tmp, "libtq.so")
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        shutil.copyfile(tmp_lib, LIB + ".tmp")
        os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
