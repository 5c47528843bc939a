"""Build of the HIP library libflint_moe.so for gfx950 (hipcc, in-tree).

The library is compiled every time ``build()`` runs; nothing is taken from
a JIT cache.  Each source is compiled to an object file in its own hipcc
process (all at once), then the objects are linked.
``-Xclang -target-feature -Xclang -packed-fp32-ops`` keeps the compiler from
emitting packed fp32 VALU instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libflint_moe.so")
SOURCES = ["repack.hip", "decode.hip", "prefill.hip", "fused.hip", "flint_b1.hip", "flint_b8.hip", "noalloc.hip", "stream.hip", "attn_prep.hip", "attn_decode.hip", "api.cpp"]
ARCH = "gfx950"
NOISE = "'-packed-fp32-ops' is not a recognized feature"


def compile_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result", "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc_command(out: str = LIB_PATH) -> list:
    """One hipcc line that compiles and links every source (reference form)."""
    return ["hipcc"] + compile_flags() + ["-shared"] + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out]


def _check(res, cmd):
    err = "\n".join(ln for ln in res.stderr.splitlines() if NOISE not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory(prefix="flint_build_") as td:
        jobs, objs = [], []
        for s in SOURCES:
            obj = os.path.join(td, os.path.splitext(s)[0] + ".o")
            cmd = ["hipcc"] + compile_flags() + ["-c", os.path.join(CSRC, s), "-o", obj]
            jobs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        errs = []
        for cmd, p in jobs:
            out, err = p.communicate()
            errs.append(_check(subprocess.CompletedProcess(cmd, p.returncode, out, err), cmd))
        link = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
        errs.append(_check(subprocess.run(link, capture_output=True, text=True), link))
    if verbose and any(e.strip() for e in errs):
        print("\n".join(e for e in errs if e.strip()), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
