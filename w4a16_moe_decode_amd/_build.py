"""Build of the HIP library libflint_moe.so for gfx950 (hipcc, in-tree).

The library is compiled every time ``build()`` runs; nothing is taken from
a JIT cache.  ``-Xclang -target-feature -Xclang -packed-fp32-ops`` keeps the
compiler from emitting packed fp32 VALU instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libflint_moe.so")
SOURCES = ["repack.hip", "decode.hip", "prefill.hip", "fused.hip", "fused_bn.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc_command(out: str = LIB_PATH) -> list:
    return (["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result", "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
            + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out])


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = hipcc_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
